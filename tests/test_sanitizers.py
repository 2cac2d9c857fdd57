"""AddressSanitizer + UndefinedBehaviorSanitizer builds of the CPU code: the
oracle (oracle/tq_oracle.c) and the host side of the C ABI (tq_host.cpp),
each driven by a harness over the shapes, edge cases and argument checks the
other tests use.  Host code only (no kernel is built or run); any memory
error, leak or undefined behaviour aborts the harness."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
       "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r.stdout


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-std=c11", *SAN, os.path.join(ROOT, "tests", "san_oracle_harness.c"),
          os.path.join(ROOT, "oracle", "tq_oracle.c"), "-o", exe, "-lm"])
    assert "oracle harness ok" in _run([exe], env=ENV, timeout=600)


@pytest.mark.skipif(not os.path.isdir("/opt/rocm/include"), reason="ROCm headers not present")
def test_host_abi_under_sanitizers(tmp_path):
    exe = str(tmp_path / "host_san")
    csrc = os.path.join(ROOT, "kv_cache_quantization_tq_amd", "csrc")
    # host code with the ROCm runtime headers (the AMD platform macro selects
    # their AMD half); the harness supplies the launchers
    _run(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
          "-I" + os.path.join(ROOT, "include"), "-I" + csrc,
          os.path.join(ROOT, "tests", "san_host_harness.cpp"), os.path.join(csrc, "tq_host.cpp"),
          "-o", exe, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"])
    assert "host harness ok" in _run([exe], env=ENV, timeout=600)
