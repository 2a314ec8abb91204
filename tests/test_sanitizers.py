"""AddressSanitizer / UndefinedBehaviorSanitizer runs of the host code, on the CPU.

Two programs are built into a temporary folder and run:

* ``tests/sanitize/oracle_driver.c`` with ``oracle/ssm_oracle.c``: every entry
  point of the C oracle, with and without its optional inputs, groups, the
  zero-order hold, empty sequences and the error returns.
* ``tests/sanitize/api_driver.cpp`` with the library's C ABI layer
  (``csrc/api.cpp``) and host stand-ins for its launches
  (``tests/sanitize/api_stubs.cpp``): every entry point through its valid
  calls and its refusals (null or overlapping pointers, bad sizes, flags,
  strides and workspaces, an allocation-free plan over its limit).

Both are host-only builds with gcc / g++ (no HIP source is compiled); any
sanitizer report aborts the program, which fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, timeout, env=None):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=timeout, env=env)
    return r.returncode, r.stdout + r.stderr


def _need(tool):
    if shutil.which(tool) is None:
        pytest.skip(f"{tool} not found")


def _check_clean(rc, out):
    assert "AddressSanitizer" not in out, out
    assert "runtime error" not in out, out
    assert "LeakSanitizer" not in out, out
    assert rc == 0, out


def test_oracle_under_sanitizers(tmp_path):
    _need("gcc")
    exe = str(tmp_path / "oracle_driver")
    rc, out = _run(["gcc", "-std=c99", *SAN, "-fopenmp",
                    "-I", os.path.join(ROOT, "oracle"),
                    os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"),
                    os.path.join(ROOT, "oracle", "ssm_oracle.c"), "-lm", "-o", exe], 300)
    assert rc == 0, out
    rc, out = _run([exe], 300, dict(ENV, OMP_NUM_THREADS="2"))
    _check_clean(rc, out)
    assert "every case ran clean" in out, out


def test_abi_layer_under_sanitizers(tmp_path):
    _need("g++")
    if not os.path.isdir("/opt/rocm/include/hip"):
        pytest.skip("HIP headers not found")
    csrc = os.path.join(ROOT, "selective_state_space_56_amd", "csrc")
    san_dir = os.path.join(ROOT, "tests", "sanitize")
    flags = ["-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
             "-I", os.path.join(ROOT, "include"), "-I", csrc]
    objs = []
    for src in (os.path.join(csrc, "api.cpp"), os.path.join(san_dir, "api_stubs.cpp"),
                os.path.join(san_dir, "api_driver.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        rc, out = _run(["g++", *flags, "-c", src, "-o", obj], 300)
        assert rc == 0, out
        objs.append(obj)
    exe = str(tmp_path / "api_driver")
    rc, out = _run(["g++", *SAN, *objs, "-o", exe], 300)
    assert rc == 0, out
    rc, out = _run([exe], 120, ENV)
    _check_clean(rc, out)
    assert "every case ran clean" in out, out
