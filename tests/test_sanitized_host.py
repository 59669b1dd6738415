"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two builds with the host compiler, each run as its own process:

* the C ABI layer of libada (``csrc/ada_api.cpp``) with host-only stand-ins
  for the kernel launchers (``tests/sanitize/launch_stubs.cpp``, which also
  check every launch description), driven by ``tests/sanitize/abi_driver.cpp``:
  every entry point through its validation, planning and dispatch paths, on
  fixed edge cases and a seeded fuzz of 20 000 argument sets;
* the CPU oracle (``oracle/ada_oracle.c``, test infrastructure) driven by
  ``tests/sanitize/oracle_driver.c`` on seeded small inputs with empty,
  negative, clamped and ragged lengths, NaN cache tails and appends outside
  the cache.

Either run fails on a sanitizer report (halt_on_error) or a failed check.
No GPU code is built or run here.
"""
import os
import shutil
import subprocess
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _run(cmd, cwd):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True, env=ENV, timeout=600)
    assert r.returncode == 0, f"{' '.join(map(str, cmd))} failed ({r.returncode}):\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r


@pytest.mark.skipif(shutil.which("g++") is None or not Path("/opt/rocm/include/hip/hip_runtime.h").exists(),
                    reason="needs g++ and the ROCm headers")
def test_abi_host_code_under_sanitizers(tmp_path):
    csrc = ROOT / "autoregressive_decode_attention_amd" / "csrc"
    exe = tmp_path / "abi_driver"
    _run(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", f"-I{ROOT / 'include'}",
          f"-I{csrc}", str(csrc / "ada_api.cpp"), str(ROOT / "tests" / "sanitize" / "launch_stubs.cpp"),
          str(ROOT / "tests" / "sanitize" / "abi_driver.cpp"), "-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib",
          "-lamdhip64", "-o", str(exe)], tmp_path)
    r = _run([str(exe)], tmp_path)
    assert "0 failures" in r.stdout, r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = tmp_path / "oracle_driver"
    _run(["gcc", "-std=c11", *SAN, str(ROOT / "oracle" / "ada_oracle.c"),
          str(ROOT / "tests" / "sanitize" / "oracle_driver.c"), "-lm", "-o", str(exe)], tmp_path)
    r = _run([str(exe)], tmp_path)
    assert "0 failures" in r.stdout, r.stdout
